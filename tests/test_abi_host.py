"""The C-ABI library on the host (no GPU): it loads, exports every entry point
include/sv.h declares, sizes workspaces, and rejects bad arguments before
launching anything.  Every call made here returns during host-side argument
validation."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# SV_ABI_LIB: another build of the same entry points (the host-sanitized one of
# test_abi_host_sanitized.py); by default the library the package loads
LIB = os.environ.get("SV_ABI_LIB") or os.path.join(ROOT, "draft_token_verification_sv_amd", "libsv.so")
HEADER = os.path.join(ROOT, "include", "sv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "sv_build", os.path.join(ROOT, "draft_token_verification_sv_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    L = ctypes.CDLL(LIB)
    L.sv_error_string.restype = ctypes.c_char_p
    L.sv_verify_attn_workspace_size.restype = ctypes.c_size_t
    L.sv_greedy_accept_workspace_size.restype = ctypes.c_size_t
    return L


class KV(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("capacity", ctypes.c_int64), ("n_seqs", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("layer_stride", ctypes.c_int64), ("scale_layer_stride", ctypes.c_int64)]


FAKE = 0x7F0000000000        # aligned, never dereferenced by the host checks


def kv(**kw):
    d = KV(dtype=1, n_kv_heads=4, head_dim=256, page_size=0, capacity=4200, n_seqs=1,
           max_pages_per_seq=0, k=FAKE, v=FAKE + 0x100000, k_scale=None, v_scale=None,
           page_table=None, layer_stride=0, scale_layer_stride=0)
    for k_, v_ in kw.items():
        setattr(d, k_, v_)
    return d


def test_exports_every_declared_symbol(lib):
    with open(HEADER) as f:
        text = f.read()
    names = set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text))
    assert {"sv_verify_attn", "sv_greedy_accept", "sv_kv_compact"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), n


def test_error_strings(lib):
    for code, text in [(0, b"ok"), (-1, b"invalid argument"), (-3, b"workspace missing or too small")]:
        assert lib.sv_error_string(code) == text
    assert lib.sv_last_hip_error() == 0


def _attn(lib, d, B=1, N=8, Hq=24, max_ctx=4096, q=FAKE, qd=1, ws=FAKE, wsb=1 << 40):
    return lib.sv_verify_attn(ctypes.byref(d) if d is not None else None, B, N, Hq,
                              ctypes.c_void_p(FAKE), max_ctx, ctypes.c_void_p(q), qd,
                              ctypes.c_void_p(FAKE), ctypes.c_float(0.0), ctypes.c_void_p(FAKE),
                              None, ctypes.c_void_p(ws), ctypes.c_size_t(wsb), None)


def test_attention_argument_checks(lib):
    assert _attn(lib, None) == -1
    assert _attn(lib, kv(head_dim=96)) == -1
    assert _attn(lib, kv(dtype=7)) == -1
    assert _attn(lib, kv(), Hq=25) == -1                   # Hq % Hkv
    assert _attn(lib, kv(), N=0) == -1
    assert _attn(lib, kv(), N=65) == -1
    assert _attn(lib, kv(capacity=4100)) == -1             # ctx + N over capacity
    assert _attn(lib, kv(n_seqs=0)) == -1
    assert _attn(lib, kv(k=FAKE + 8)) == -1                # misaligned
    assert _attn(lib, kv(), q=0) == -1
    assert _attn(lib, kv(), qd=2) == -1
    assert _attn(lib, kv(dtype=2)) == -1                   # 4-bit without scales
    assert _attn(lib, kv(dtype=0), qd=1) == -2             # bf16 q over an fp32 cache
    assert _attn(lib, kv(page_size=12, page_table=FAKE, max_pages_per_seq=400)) == -1
    assert _attn(lib, kv(page_size=16, page_table=FAKE, max_pages_per_seq=256)) == -1   # 4096 < ctx+N
    assert _attn(lib, kv(), ws=0) == -3
    assert _attn(lib, kv(), wsb=1024) == -3
    assert _attn(lib, kv(n_seqs=1025), B=1025, max_ctx=64) == -2   # batch over 1024
    assert _attn(lib, kv(n_seqs=1024), B=1024, max_ctx=64, wsb=1024) == -3


def test_attention_workspace_size(lib):
    d = kv()
    n = lib.sv_verify_attn_workspace_size(ctypes.byref(d), 1, 8, 24, 4096)
    # partials (O and m,l) of 48 rows x 256 dims per (KV head, split): at least one split per head
    assert n >= 4 * 48 * (256 + 2) * 4 and n % 256 == 0
    assert lib.sv_verify_attn_workspace_size(ctypes.byref(d), 1, 8, 25, 4096) == 0
    big = lib.sv_verify_attn_workspace_size(ctypes.byref(kv(capacity=200000)), 1, 8, 24, 131072)
    assert big >= n
    # a batch: partial slots for at least two units per (sequence, KV head)
    # plus the 16-byte per-sequence schedule record
    nb = lib.sv_verify_attn_workspace_size(ctypes.byref(kv(n_seqs=64)), 64, 8, 24, 4096)
    assert nb >= 2 * 64 * 4 * 48 * (256 + 2) * 4 + 64 * 16 and nb % 256 == 0


def test_split_plan_keeps_the_grid_for_a_short_remainder(lib):
    """One sequence over a 4-bit cache (24/4 heads, 16 rows, head dim 256):
    a key range 16 keys over 64 * 2048 keeps 64 splits per KV head (the last
    split takes the 16), so its partial slots equal those of exactly 64 * 2048
    keys; the plan that rounds every split up to the 128-key stage would have
    61 splits (fewer slots)."""
    d = kv(dtype=2, k_scale=FAKE + 0x200000, v_scale=FAKE + 0x300000, capacity=140000)
    exact = lib.sv_verify_attn_workspace_size(ctypes.byref(d), 1, 16, 24, 131072 - 16)
    over = lib.sv_verify_attn_workspace_size(ctypes.byref(d), 1, 16, 24, 131072)
    assert exact > 0 and over == exact
    per_split = 4 * 96 * (256 + 2) * 4          # O and (m, l) of 96 rows, four KV heads
    assert over >= 64 * per_split and over < 65 * per_split


def test_accept_checks_and_workspace(lib):
    n = lib.sv_greedy_accept_workspace_size(1, 8, 151936)
    # one 64-bit key per row, one counter per sequence
    assert n == 2 * 256
    assert lib.sv_greedy_accept_workspace_size(8, 64, 151936) == 4096 + 256
    P = ctypes.c_void_p(FAKE)

    def call(B=1, N=8, V=151936, ld=1, ws=FAKE, wsb=1 << 30):
        return lib.sv_greedy_accept(B, N, V, P, ld, P, P, P, P, P, None, ctypes.c_void_p(ws),
                                    ctypes.c_size_t(wsb), None)
    assert call(N=0) == -1 and call(N=65) == -1 and call(V=0) == -1 and call(ld=2) == -1
    assert call(ws=0) == -3 and call(wsb=16) == -3
    assert lib.sv_greedy_accept(1, 8, 100, None, 1, P, P, P, P, P, None, P, ctypes.c_size_t(1 << 20), None) == -1


def test_compact_checks(lib):
    P = ctypes.c_void_p(FAKE)

    def call(d, L=1, B=1, N=8, max_ctx=4096):
        return lib.sv_kv_compact(ctypes.byref(d), L, B, N, P, max_ctx, P, P, None, None)
    assert call(kv(), L=0) == -1
    assert call(kv(), L=3) == -1                            # several layers need a layer stride
    assert call(kv(layer_stride=24)) == -1                  # stride not a multiple of 16
    assert call(kv(), N=70) == -1
    assert call(kv(capacity=10)) == -1


def test_accept_compact_checks(lib):
    P = ctypes.c_void_p(FAKE)

    def call(d=None, B=1, N=8, V=151936, L=1, ld=1, ctx=FAKE, ws=FAKE, wsb=1 << 30):
        d = kv() if d is None else d
        return lib.sv_greedy_accept_compact(B, N, V, P, ld, P, P, P, P, P, None, ctypes.byref(d), L,
                                            ctypes.c_void_p(ctx), 4096, None, ctypes.c_void_p(ws),
                                            ctypes.c_size_t(wsb), None)
    # the checks of both calls apply
    assert call(N=0) == -1 and call(N=65) == -1 and call(V=0) == -1 and call(ld=2) == -1
    assert call(ws=0) == -3 and call(wsb=16) == -3
    assert call(L=0) == -1 and call(L=3) == -1 and call(ctx=0) == -1
    assert call(d=kv(capacity=10)) == -1 and call(d=kv(layer_stride=24)) == -1


def test_kv_append_checks(lib):
    P = ctypes.c_void_p(FAKE)

    def call(d=None, B=1, n=8, ctx=FAKE, k=FAKE, src=1, max_ctx=4096):
        d = kv() if d is None else d
        return lib.sv_kv_append(ctypes.byref(d), B, n, ctypes.c_void_p(ctx), max_ctx, ctypes.c_void_p(k), P,
                                src, None)
    assert call(n=0) == -1 and call(n=65) == -1 and call(B=0) == -1
    assert call(src=2) == -1 and call(src=7) == -1          # sources are fp32 or bf16
    assert call(ctx=0) == -1 and call(k=0) == -1 and call(k=FAKE + 8) == -1
    assert call(d=kv(capacity=4100)) == -1                   # 4096 + 8 rows do not fit


def test_window_checks(lib):
    lib.sv_verify_attn_window_workspace_size.restype = ctypes.c_size_t
    d = kv()
    full = lib.sv_verify_attn_workspace_size(ctypes.byref(d), 1, 8, 24, 4096)
    assert lib.sv_verify_attn_window_workspace_size(ctypes.byref(d), 1, 8, 24, 4096, 0) == full
    assert lib.sv_verify_attn_window_workspace_size(ctypes.byref(d), 1, 8, 24, 4096, 2048) > 0
    assert lib.sv_verify_attn_window_workspace_size(ctypes.byref(d), 1, 8, 24, 4096, 7) == 0   # < N
    assert lib.sv_verify_attn_window_workspace_size(ctypes.byref(d), 1, 8, 24, 4096, -1) == 0
    P = ctypes.c_void_p(FAKE)

    def call(w):
        return lib.sv_verify_attn_window(ctypes.byref(d), 1, 8, 24, P, 4096, P, 1, P, ctypes.c_float(0.0), w,
                                         P, None, P, ctypes.c_size_t(1 << 30), None)
    assert call(7) == -1 and call(-5) == -1


def test_sample_accept_checks(lib):
    P = ctypes.c_void_p(FAKE)

    def call(T=0.8, g=FAKE, N=8, ws=FAKE):
        return lib.sv_sample_accept(1, N, 151936, P, 1, ctypes.c_void_p(g), ctypes.c_float(T), P, P, P, P, P,
                                    None, ctypes.c_void_p(ws), ctypes.c_size_t(1 << 30), None)
    assert call(T=0.0) == -1 and call(T=-1.0) == -1 and call(T=float("inf")) == -1 and call(T=float("nan")) == -1
    assert call(g=0) == -1 and call(g=FAKE + 2) == -1
    assert call(N=0) == -1 and call(ws=0) == -3

    def topk(k, T=0.8, g=FAKE):
        return lib.sv_sample_accept_topk(1, 8, 151936, P, 1, ctypes.c_void_p(g), ctypes.c_float(T), k, P, P, P, P,
                                         P, None, P, ctypes.c_size_t(1 << 30), None)
    assert topk(1025) == -2 and topk(151935) == -2            # 1 <= k <= 1024 on the top-k kernel
    assert topk(50, T=0.0) == -1 and topk(50, g=0) == -1 and topk(0, g=0) == -1


def test_recurrent_checks(lib):
    P = ctypes.c_void_p(FAKE)
    I64 = ctypes.c_int64

    def conv(B=1, N=22, C=10240, K=4, x=FAKE, dt=1, act=1, bias=None):
        return lib.sv_ssm_conv_tree(B, N, C, K, ctypes.c_void_p(x), P, dt, P, bias, None, act, P, None)
    assert conv(N=0) == -1 and conv(N=65) == -1 and conv(B=0) == -1
    assert conv(C=10) == -1 and conv(K=1) == -1 and conv(K=5) == -1
    assert conv(dt=2) == -1 and conv(act=2) == -1 and conv(x=0) == -1 and conv(x=FAKE + 8) == -1
    assert conv(bias=ctypes.c_void_p(FAKE + 4)) == -1

    def delta(N=22, Hk=16, Hv=48, Dk=128, Dv=128, qs=0, vs=0, dt=1, sdt=3, g=FAKE, scale=0.0, q=FAKE, sched=0):
        return lib.sv_gated_delta_net_tree(1, N, Hk, Hv, Dk, Dv, ctypes.c_void_p(q), P, P, I64(qs), I64(vs), dt,
                                           ctypes.c_void_p(g), P, P, None, ctypes.c_void_p(sched),
                                           ctypes.c_float(scale), P, P, sdt, None)
    assert delta(N=65) == -1 and delta(Hv=40) == -1            # value heads a multiple of key heads
    assert delta(Dk=256) == -2 and delta(Dk=96) == -2          # key dims 64 and 128
    assert delta(Dv=48) == -1 and delta(dt=2) == -1 and delta(sdt=1) == -1
    assert delta(qs=2048 + 4) == -1 and delta(qs=1024) == -1 and delta(vs=6000) == -1
    assert delta(g=0) == -1 and delta(q=FAKE + 8) == -1 and delta(scale=float("nan")) == -1
    assert delta(sched=FAKE + 2) == -1
    assert lib.sv_tree_schedule(1, 65, P, P, None) == -1 and lib.sv_tree_schedule(1, 22, None, P, None) == -1

    def commit(N=22, K=4, sdt=3, path=FAKE, Dk=128):
        return lib.sv_recurrent_commit(1, N, 48, Dk, 128, P, sdt, P, 10240, K, P, P, 1, ctypes.c_void_p(path), P,
                                       None)
    assert commit(N=0) == -1 and commit(K=5) == -1 and commit(sdt=2) == -1
    assert commit(path=0) == -1 and commit(Dk=32) == -1


class Tuning(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("attn_target_wgs", "attn_rowblocks", "attn_posgroups",
                                              "attn_occupancy", "attn_q4_kernel", "argmax_chunk")]


def test_tuning_per_call(lib):
    """Tuning travels with the call: out-of-range fields are rejected before
    anything is launched, a null or all-zero tuning is the default plan, and
    nothing persists from one call to the next."""
    lib.sv_verify_attn_tuned_workspace_size.restype = ctypes.c_size_t
    d = kv()
    base = lib.sv_verify_attn_workspace_size(ctypes.byref(d), 1, 8, 24, 4096)
    assert base > 0

    def ws(**f):
        t = Tuning(**f)
        return lib.sv_verify_attn_tuned_workspace_size(ctypes.byref(d), 1, 8, 24, 4096, 0, ctypes.byref(t))
    assert lib.sv_verify_attn_tuned_workspace_size(ctypes.byref(d), 1, 8, 24, 4096, 0, None) == base
    assert ws() == base
    assert ws(attn_posgroups=3) == 0 and ws(attn_occupancy=3) == 0 and ws(attn_q4_kernel=4) == 0
    assert ws(attn_target_wgs=-1) == 0 and ws(attn_rowblocks=-2) == 0 and ws(argmax_chunk=12) == 0
    more = ws(attn_target_wgs=4096)                 # more splits, more partials
    assert more > base
    assert lib.sv_verify_attn_workspace_size(ctypes.byref(d), 1, 8, 24, 4096) == base   # no state kept

    P = ctypes.c_void_p(FAKE)
    bad = Tuning(attn_posgroups=3)
    rc = lib.sv_verify_attn_tuned(ctypes.byref(d), 1, 8, 24, P, 4096, P, 1, P, ctypes.c_float(0.0), 0,
                                  ctypes.byref(bad), P, None, P, ctypes.c_size_t(1 << 30), None)
    assert rc == -1
    small = Tuning(attn_target_wgs=4096)          # needs more than the default workspace
    rc = lib.sv_verify_attn_tuned(ctypes.byref(d), 1, 8, 24, P, 4096, P, 1, P, ctypes.c_float(0.0), 0,
                                  ctypes.byref(small), P, None, P, ctypes.c_size_t(base), None)
    assert rc == -3
    chunk = Tuning(argmax_chunk=12)
    rc = lib.sv_greedy_accept_tuned(1, 8, 151936, P, 1, P, P, P, P, P, None, ctypes.byref(chunk), P,
                                    ctypes.c_size_t(1 << 20), None)
    assert rc == -1
    rc = lib.sv_greedy_accept_tuned(0, 8, 151936, P, 1, P, P, P, P, P, None, None, P, ctypes.c_size_t(1 << 20),
                                    None)
    assert rc == -1


def _debug_lib():
    path = os.path.join(ROOT, "draft_token_verification_sv_amd", "libsv_debug.so")
    if not os.path.exists(path):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "sv_build", os.path.join(ROOT, "draft_token_verification_sv_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(debug=True)
    return ctypes.CDLL(path)


def test_check_device_errors_host_side(lib):
    """sv_check_device_errors: the release library records nothing and returns
    0 without touching a device; the SV_DEBUG library exports the same entry
    points and, with no GPU to read the word from, reports SV_EHIP (the HIP
    error kept for sv_last_hip_error)."""
    assert lib.sv_check_device_errors(None) == 0
    dbg = _debug_lib()
    with open(HEADER) as f:
        names = set(re.findall(r"\b(sv_[a-z_]+)\s*\(", f.read()))
    for n in sorted(names):
        assert hasattr(dbg, n), n
    import torch
    if torch.cuda.is_available():
        assert dbg.sv_check_device_errors(None) >= 0
    else:
        assert dbg.sv_check_device_errors(None) == -4
        assert dbg.sv_last_hip_error() != 0


def test_noalloc_rejects_large_plans_on_the_host(lib):
    """sv_verify_attn_noalloc: a plan whose split partials exceed the static
    32 MiB buffer (64 paged sequences of 30K keys, 32/8 heads, dim 128) returns
    SV_EWORKSPACE before any device call; bad arguments return SV_EINVAL."""
    lib.sv_verify_attn_workspace_size.restype = ctypes.c_size_t
    d = kv(dtype=1, n_kv_heads=8, head_dim=128, page_size=16, capacity=200000, n_seqs=0,
           max_pages_per_seq=(30000 + 16 + 15) // 16, page_table=FAKE + 0x200000)
    assert lib.sv_verify_attn_workspace_size(ctypes.byref(d), 64, 16, 32, 30000) > 32 << 20
    P = ctypes.c_void_p(FAKE)
    assert lib.sv_verify_attn_noalloc(ctypes.byref(d), 64, 16, 32, P, 30000, P, 1, P, ctypes.c_float(0.0), 0, P,
                                      None, None) == -3
    assert lib.sv_verify_attn_noalloc(ctypes.byref(d), 64, 0, 32, P, 30000, P, 1, P, ctypes.c_float(0.0), 0, P,
                                      None, None) == -1
    assert lib.sv_verify_attn_noalloc(ctypes.byref(d), 64, 16, 32, P, 30000, P, 1, P, ctypes.c_float(0.0), 8, P,
                                      None, None) == -1              # window below N
