"""Benchmark of one verify step on one MI355X.

A step is the whole verify path for one layer over one batch of seeded
synthetic inputs already resident in HBM: ``sv_verify_attn`` (tree/chain
masked GQA attention over the KV cache), then ``sv_greedy_accept_compact``
(vocab argmax + acceptance walk, then in-place KV compaction of the accepted
rows, in one launch; the separate ``sv_greedy_accept`` / ``sv_kv_compact``
calls are timed too, in ``breakdown_us``).  Inputs rotate
over enough device copies (>= 1 GiB) that the 256 MB Infinity Cache cannot
serve the KV cache from one step to the next.

Prints one JSON line.  ``value`` is verified draft tokens per second
(sum over sequences of N - 1 draft rows, per step time).  ``roofline``
reports the verify-attention call (split kernel + merge kernel), timed with
HIP events on the launch stream around a graph replay of `steps` calls
against the 8 TB/s HBM peak, using the algorithmic bytes of the call: every KV
row of the key range read once, plus q, out and lse.  ``cpu_baseline`` times
the fp64 CPU oracle on a bounded sample of the same workload.
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
METRIC = "verified draft tokens/s per verify step + achieved HBM GB/s (% of MI355X peak)"
WORKLOADS = {"C1": "C1", "C2": "C2", "C3": "C3", "C4": "C4", "C5": "C5"}
DEFAULT_CONFIG = "C2"        # chain verify, GQA 24/4, head dim 256, 4096 cached tokens


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


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_token_verification_sv_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, per_launch_bytes):
    """HBM bytes per call of the workload's dominant kernel (attention, or the
    tree recurrence) from the committed rocprofv3 counter runs, if they were
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "attn_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(workload)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_call")


def _blas_threads():
    """Threads numpy's BLAS may use (the oracle's only parallel part)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def cpu_baseline(cfg_key, seconds):
    """The oracle (unchanged) on a sample of the same workload: whole verify
    steps on the host cores, repeated for about `seconds`."""
    import oracle
    import workloads
    cfg = workloads.CONFIGS[cfg_key]
    case = workloads.make_case(cfg, seed=1)
    lg = case.logits.astype(np.float64) if cfg.logits_dtype == "f32" else oracle.widen_bf16(case.logits)
    steps = 0
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
    return {"value": drafts * steps / dt, "unit": "verified draft tokens/s", "cores": _blas_threads(),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{steps} whole verify steps of the {cfg.name} workload (attention, argmax + walk, "
                      f"compaction) in {dt:.1f} s, fp64 numpy"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate-bytes", type=float, default=1.1 * 2 ** 30)
    ap.add_argument("--target-wgs", type=int, default=0, help="attention grid target (0: library default)")
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
    import workloads
    import draft_token_verification_sv_amd as sv

    if args.target_wgs:
        sv.set_option(sv.SV_OPT_ATTN_TARGET_WGS, args.target_wgs)
    cfg = workloads.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    case = workloads.make_case(cfg, seed=1)

    def up(x, kind):
        x = np.ascontiguousarray(x)
        if kind == "bf16":
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        if kind == "u16":
            return torch.from_numpy(x.view(np.int16)).to(dev)
        return torch.from_numpy(x).to(dev)

    qk = "bf16" if cfg.q_dtype == "bf16" else "f32"
    base = {
        "q": up(case.q, qk),
        "logits": up(case.logits, "bf16" if cfg.logits_dtype == "bf16" else "f32"),
    }
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
    ws_a = torch.empty(sv.verify_attn_workspace_size(kvs[0], B, N, Hq, max_ctx, window=args.window),
                       dtype=torch.uint8, device=dev)
    ws_g = torch.zeros(sv.greedy_accept_workspace_size(B, N, cfg.vocab), dtype=torch.uint8, device=dev)

    def attn(i):
        c, kv = copies[i % n_copies], kvs[i % n_copies]
        sv.verify_attn(kv, c["q"], ctx, parent, max_ctx, out=outs[i & 1], lse=lse, workspace=ws_a,
                       window=args.window)

    def accept(i):
        sv.greedy_accept(copies[i % n_copies]["logits"], drafts, parent, workspace=ws_g,
                         outputs=(acc, path, tok, None))

    def compact(i):
        sv.kv_compact(kvs[i % n_copies], ctx, max_ctx, path, acc, new_lens=new_lens)

    # the verify block's K/V rows written into the cache (timed separately)
    src_kind = "bf16" if cfg.q_dtype == "bf16" else "f32"
    rng_new = np.random.default_rng(977)
    new_rows = [up((rng_new.standard_normal((B, N, cfg.n_kv_heads, D)) * 0.5).astype(np.float32)
                   if src_kind == "f32" else
                   workloads.bf16_bits((rng_new.standard_normal((B, N, cfg.n_kv_heads, D)) * 0.5).astype(np.float32)),
                   src_kind) for _ in range(2)]

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

    def accept_compact(i):
        sv.greedy_accept_compact(copies[i % n_copies]["logits"], drafts, parent, kvs[i % n_copies], ctx, max_ctx,
                                 workspace=ws_g, outputs=(acc, path, tok, None), new_lens=new_lens)

    # one verify step: attention, then acceptance and compaction in one launch
    # (the separate calls are timed below for the breakdown)
    def step(i):
        attn(i)
        accept_compact(i)

    # warm-up: eager steps (first launches, code objects, caches)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed work is replayed from HIP graphs (the launch path a serving loop
    # uses); each graph holds exactly `steps` consecutive calls over the rotation.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.steps):
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

    g_step = capture(step)
    total_ms = timed(g_step)
    g_attn = capture(attn)
    attn_total_ms = timed(g_attn)
    g_acc = capture(accept)
    accept_us = timed(g_acc) / args.steps * 1e3
    g_cmp = capture(compact)
    compact_us = timed(g_cmp) / args.steps * 1e3
    g_ac = capture(accept_compact)
    accept_compact_us = timed(g_ac) / args.steps * 1e3
    g_smp = capture(sample)
    sample_us = timed(g_smp) / args.steps * 1e3
    g_stk = capture(sample_topk)
    sample_topk_us = timed(g_stk) / args.steps * 1e3
    g_app = capture(append)                 # last: it rewrites the draft rows of the rotated caches
    append_us = timed(g_app) / args.steps * 1e3
    attn_ms = np.array([attn_total_ms / args.steps])

    ms_per_step = total_ms / args.steps
    drafts_per_step = B * (N - 1)
    value = drafts_per_step / (ms_per_step / 1e3)
    attn_bytes = attn_algorithmic_bytes(cfg, case.ctx_lens, args.window)
    attn_us = float(np.mean(attn_ms) * 1e3)
    achieved = attn_bytes / (attn_us * 1e-6) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.q_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": D, "n_nodes": N, "tree": cfg.tree, "kv": cfg.kv_dtype,
                   "kv_layout": "paged16" if cfg.paged else "contiguous",
                   "ctx": int(cfg.ctx) if not cfg.ctx_hi else [int(cfg.ctx), int(cfg.ctx_hi)],
                   "vocab": cfg.vocab, "rotation_copies": n_copies, "window": args.window},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if args.window else measured_traffic(cfg.name, attn_bytes),
                     "kernel": "sv_verify_attn (split + merge kernels)",
                     "algorithmic_bytes": int(attn_bytes)},
        "breakdown_us": {"verify_attn": round(attn_us, 2), "greedy_accept": round(accept_us, 2),
                         "kv_compact": round(compact_us, 2), "greedy_accept_compact": round(accept_compact_us, 2),
                         "kv_append (not in the step)": round(append_us, 2),
                         "sample_accept T=0.8 (not in the step)": round(sample_us, 2),
                         "sample_accept_topk k=50 T=0.8 (not in the step)": round(sample_topk_us, 2)},
        "accepted_tokens_per_step": None,
    }
    if args.recurrent != "none":
        rec["recurrent"] = recurrent_bench(sv, dev, args.recurrent, args.steps, args.rotate_bytes, capture, timed)
        if not args.no_cpu_baseline:
            rec["recurrent"]["cpu_baseline"] = recurrent_cpu_baseline(args.recurrent, min(5.0, args.cpu_seconds))
    a_host = acc.cpu().numpy()
    rec["accepted_tokens_per_step"] = int(np.sum(a_host + 1))
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.config, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
