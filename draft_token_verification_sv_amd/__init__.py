"""Python binding of the gfx950 verify-step library (``libsv.so``).

Argument marshalling only: every step of the verify path runs in the HIP
kernels behind the C ABI of ``include/sv.h``.  PyTorch supplies device memory
and the current stream.  Importing this package loads the library and raises
if it has not been built; there is no fallback implementation.  With the
environment variable ``SV_DEBUG=1`` it loads ``libsv_debug.so`` (kernels that
record broken device-side inputs; read them with ``check_device_errors``).

    kv = KVCache.contiguous(k, v)                 # [B, Hkv, cap, D] bf16/fp32
    out, lse = verify_attn(kv, q, ctx_lens, parent, max_ctx)
    acc, path, tokens, am = greedy_accept(logits, draft_ids, parent)
    new_lens = kv_compact(kv, ctx_lens, max_ctx, path, acc)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "SV_F32", "SV_BF16", "SV_Q4", "SVError", "KVCache", "lib", "library_path",
    "verify_attn", "verify_attn_workspace_size", "greedy_accept", "greedy_accept_workspace_size",
    "kv_compact", "greedy_accept_compact", "kv_append", "sample_accept", "SV_F16", "TUNING_FIELDS",
    "check_device_errors", "SV_DEVERR_PARENT", "SV_DEVERR_PAGE", "SV_DEVERR_CTX", "SV_DEVERR_PATH",
    "ssm_conv_tree", "gated_delta_net_tree", "recurrent_commit", "tree_schedule", "debug_build",
    "verify_attn_noalloc", "NOALLOC_SCRATCH_BYTES",
]

SV_F32, SV_BF16, SV_Q4, SV_F16 = 0, 1, 2, 3
SV_DEVERR_PARENT, SV_DEVERR_PAGE, SV_DEVERR_CTX, SV_DEVERR_PATH = 1, 2, 4, 8

debug_build = os.environ.get("SV_DEBUG", "") not in ("", "0")
library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                            "libsv_debug.so" if debug_build else "libsv.so")
if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is missing: build it with `python draft_token_verification_sv_amd/build.py"
        f"{' --debug' if debug_build else ''}` (there is no CPU fallback)")
lib = ctypes.CDLL(library_path)


class _KvDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("n_seqs", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("layer_stride", ctypes.c_int64),
        ("scale_layer_stride", ctypes.c_int64),
    ]


# sv_tuning: per-call launch tuning (0 = the library's choice for every field)
TUNING_FIELDS = ("attn_target_wgs", "attn_rowblocks", "attn_posgroups", "attn_occupancy", "attn_q4_kernel",
                 "argmax_chunk")


class _Tuning(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in TUNING_FIELDS]


def _tuning(tuning) -> Optional[_Tuning]:
    """A dict of sv_tuning fields (``attn_q4_kernel`` may also be
    "cooperative" (the four-wave cooperative kernel), "pipelined" or "wide"
    (the eight-wave cooperative kernel, also the default)) -> the struct, or
    None."""
    if not tuning:
        return None
    t = _Tuning()
    for key, val in tuning.items():
        if key not in TUNING_FIELDS:
            raise ValueError(f"unknown tuning field {key!r}")
        if key == "attn_q4_kernel" and isinstance(val, str):
            val = {"cooperative": 1, "pipelined": 2, "wide": 3}[val]
        setattr(t, key, int(val))
    return t


def _tref(t: Optional[_Tuning]):
    return None if t is None else ctypes.byref(t)


_P = ctypes.c_void_p
_I = ctypes.c_int
lib.sv_verify_attn_workspace_size.restype = ctypes.c_size_t
lib.sv_verify_attn_workspace_size.argtypes = [ctypes.POINTER(_KvDesc), _I, _I, _I, _I]
lib.sv_verify_attn.restype = _I
lib.sv_verify_attn.argtypes = [ctypes.POINTER(_KvDesc), _I, _I, _I, _P, _I, _P, _I, _P,
                               ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]
lib.sv_verify_attn_window_workspace_size.restype = ctypes.c_size_t
lib.sv_verify_attn_window_workspace_size.argtypes = [ctypes.POINTER(_KvDesc), _I, _I, _I, _I, _I]
lib.sv_verify_attn_window.restype = _I
lib.sv_verify_attn_window.argtypes = [ctypes.POINTER(_KvDesc), _I, _I, _I, _P, _I, _P, _I, _P,
                                      ctypes.c_float, _I, _P, _P, _P, ctypes.c_size_t, _P]
lib.sv_greedy_accept_workspace_size.restype = ctypes.c_size_t
lib.sv_greedy_accept_workspace_size.argtypes = [_I, _I, _I]
lib.sv_greedy_accept.restype = _I
lib.sv_greedy_accept.argtypes = [_I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.sv_kv_compact.restype = _I
lib.sv_kv_compact.argtypes = [ctypes.POINTER(_KvDesc), _I, _I, _I, _P, _I, _P, _P, _P, _P]
lib.sv_sample_accept.restype = _I
lib.sv_sample_accept.argtypes = [_I, _I, _I, _P, _I, _P, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P,
                                 ctypes.c_size_t, _P]
lib.sv_kv_append.restype = _I
lib.sv_kv_append.argtypes = [ctypes.POINTER(_KvDesc), _I, _I, _P, _I, _P, _P, _I, _P]
lib.sv_greedy_accept_compact.restype = _I
lib.sv_greedy_accept_compact.argtypes = [_I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P,
                                         ctypes.POINTER(_KvDesc), _I, _P, _I, _P, _P, ctypes.c_size_t, _P]
lib.sv_sample_accept_topk.restype = _I
lib.sv_sample_accept_topk.argtypes = [_I, _I, _I, _P, _I, _P, ctypes.c_float, _I, _P, _P, _P, _P, _P, _P, _P,
                                      ctypes.c_size_t, _P]
lib.sv_ssm_conv_tree.restype = _I
lib.sv_ssm_conv_tree.argtypes = [_I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _I, _P, _P]
lib.sv_gated_delta_net_tree.restype = _I
lib.sv_gated_delta_net_tree.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, ctypes.c_int64, ctypes.c_int64, _I,
                                        _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _I, _P]
lib.sv_tree_schedule.restype = _I
lib.sv_tree_schedule.argtypes = [_I, _I, _P, _P, _P]
lib.sv_recurrent_commit.restype = _I
lib.sv_recurrent_commit.argtypes = [_I, _I, _I, _I, _I, _P, _I, _P, _I, _I, _P, _P, _I, _P, _P, _P]
lib.sv_error_string.restype = ctypes.c_char_p
lib.sv_error_string.argtypes = [_I]
lib.sv_last_hip_error.restype = _I
lib.sv_verify_attn_tuned_workspace_size.restype = ctypes.c_size_t
lib.sv_verify_attn_tuned_workspace_size.argtypes = [ctypes.POINTER(_KvDesc), _I, _I, _I, _I, _I,
                                                    ctypes.POINTER(_Tuning)]
lib.sv_verify_attn_tuned.restype = _I
lib.sv_verify_attn_tuned.argtypes = [ctypes.POINTER(_KvDesc), _I, _I, _I, _P, _I, _P, _I, _P,
                                     ctypes.c_float, _I, ctypes.POINTER(_Tuning), _P, _P, _P, ctypes.c_size_t, _P]
lib.sv_greedy_accept_tuned.restype = _I
lib.sv_greedy_accept_tuned.argtypes = [_I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Tuning), _P,
                                       ctypes.c_size_t, _P]
lib.sv_verify_attn_noalloc.restype = _I
lib.sv_verify_attn_noalloc.argtypes = [ctypes.POINTER(_KvDesc), _I, _I, _I, _P, _I, _P, _I, _P, ctypes.c_float, _I,
                                       _P, _P, _P]
NOALLOC_SCRATCH_BYTES = 32 << 20
lib.sv_check_device_errors.restype = _I
lib.sv_check_device_errors.argtypes = [_P]


class SVError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = lib.sv_error_string(code).decode()
        if code == -4:
            msg += f" (hipError {lib.sv_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{code}]")
        self.code = code


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise SVError(rc, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


@dataclass
class KVCache:
    """Device KV cache views (no copies).

    Contiguous: ``k``/``v`` are ``[B, Hkv, cap, D]`` (fp32/bf16) or
    ``[B, Hkv, cap, D/2]`` uint8 4-bit codes with ``k_scale``/``v_scale``
    ``[B, Hkv, cap, D/32]`` (fp16, as int16/uint16/float16).  Paged: the same
    with the leading two axes ``[pages, Hkv, page_size, ...]`` and a
    ``page_table`` int32 ``[B, max_pages]``.  An extra leading layer axis makes
    a multi-layer cache (``kv_compact`` walks every layer; attention reads
    layer ``layer``).
    """
    k: torch.Tensor
    v: torch.Tensor
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    page_table: Optional[torch.Tensor] = None
    head_dim: int = 0

    @property
    def q4(self) -> bool:
        return self.k.dtype == torch.uint8

    @property
    def n_layers(self) -> int:
        return self.k.shape[0] if self.k.dim() == 5 else 1

    def desc(self, layer: int = 0) -> _KvDesc:
        k, v = self.k, self.v
        for t in (k, v, self.k_scale, self.v_scale, self.page_table):
            if t is not None and not t.is_contiguous():
                raise ValueError("KV tensors must be contiguous")
        multi = k.dim() == 5
        kl = k[layer] if multi else k
        vl = v[layer] if multi else v
        d = _KvDesc()
        if self.q4:
            if self.k_scale is None or self.v_scale is None:
                raise ValueError("4-bit cache needs k_scale and v_scale")
            d.dtype = SV_Q4
            d.head_dim = kl.shape[-1] * 2
            ks = self.k_scale[layer] if multi else self.k_scale
            vs = self.v_scale[layer] if multi else self.v_scale
            d.k_scale, d.v_scale = ks.data_ptr(), vs.data_ptr()
            d.scale_layer_stride = (self.k_scale.stride(0) * self.k_scale.element_size()) if multi else 0
        else:
            d.dtype = _dtype_code(kl)
            d.head_dim = kl.shape[-1]
            d.k_scale = d.v_scale = None
            d.scale_layer_stride = 0
        if self.head_dim and self.head_dim != d.head_dim:
            raise ValueError("head_dim mismatch")
        d.n_kv_heads = kl.shape[1]
        d.k, d.v = kl.data_ptr(), vl.data_ptr()
        d.layer_stride = (k.stride(0) * k.element_size()) if multi else 0
        if self.page_table is None:
            d.page_size = 0
            d.capacity = kl.shape[2]
            d.n_seqs = kl.shape[0]
            d.max_pages_per_seq = 0
            d.page_table = None
        else:
            if self.page_table.dtype != torch.int32:
                raise TypeError("page_table must be int32")
            d.page_size = kl.shape[2]
            d.capacity = kl.shape[0]
            d.n_seqs = 0
            d.max_pages_per_seq = self.page_table.shape[1]
            d.page_table = self.page_table.data_ptr()
        return d

    @classmethod
    def contiguous(cls, k, v, k_scale=None, v_scale=None):
        return cls(k=k, v=v, k_scale=k_scale, v_scale=v_scale)

    @classmethod
    def paged(cls, k, v, page_table, k_scale=None, v_scale=None):
        return cls(k=k, v=v, k_scale=k_scale, v_scale=v_scale, page_table=page_table)


# Default workspaces, one per (kind, device, stream): a workspace serves one
# stream at a time, and each is allocated while its stream is current, so the
# caching allocator orders its reuse on that same stream.
_ws_cache: dict = {}


def _ws_key(kind: str, dev: torch.device) -> tuple:
    return (kind, torch.device(dev).index, _stream(dev))


def _workspace(kind: str, dev: torch.device, nbytes: int, zero: bool) -> torch.Tensor:
    key = _ws_key(kind, dev)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        size = max(nbytes, 256)
        buf = (torch.zeros if zero else torch.empty)(size, dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


def _drop_workspace(kind: str, dev: torch.device) -> None:
    """Forget a default workspace after a failed call (an acceptance workspace
    must be all zeros on entry; a failed call may not have left it so)."""
    _ws_cache.pop(_ws_key(kind, dev), None)


def _check_ws(rc: int, where: str, kind: str, dev: torch.device, default_ws: bool) -> None:
    if rc != 0 and default_ws:
        _drop_workspace(kind, dev)
    _check(rc, where)


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
        raise TypeError(f"{name} must be a contiguous int32 device tensor")
    return t


def verify_attn_workspace_size(kv: KVCache, batch: int, n_nodes: int, n_q_heads: int, max_ctx: int,
                               window: int = 0, tuning: Optional[dict] = None) -> int:
    d = kv.desc()
    t = _tuning(tuning)
    if t is not None:
        return int(lib.sv_verify_attn_tuned_workspace_size(ctypes.byref(d), batch, n_nodes, n_q_heads, max_ctx,
                                                           window, _tref(t)))
    if window:
        return int(lib.sv_verify_attn_window_workspace_size(ctypes.byref(d), batch, n_nodes, n_q_heads, max_ctx,
                                                            window))
    return int(lib.sv_verify_attn_workspace_size(ctypes.byref(d), batch, n_nodes, n_q_heads, max_ctx))


def verify_attn(kv: KVCache, q: torch.Tensor, ctx_lens: torch.Tensor, parent: torch.Tensor,
                max_ctx: int, sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                workspace: Optional[torch.Tensor] = None, layer: int = 0, window: int = 0,
                tuning: Optional[dict] = None):
    """Masked GQA attention of the verify rows.  ``q`` ``[B, N, Hq, D]``.

    ``window`` > 0: only the last ``window`` key rows of each sequence.
    ``tuning``: sv_tuning fields for this call (see ``TUNING_FIELDS``)."""
    if q.dim() != 4 or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q must be a contiguous [B, N, Hq, D] device tensor")
    B, N, Hq, D = q.shape
    _i32(ctx_lens, "ctx_lens")
    _i32(parent, "parent")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=q.device)
    d = kv.desc(layer)
    t = _tuning(tuning)
    default_ws = workspace is None
    if default_ws:
        need = int(lib.sv_verify_attn_tuned_workspace_size(ctypes.byref(d), B, N, Hq, int(max_ctx), int(window),
                                                           _tref(t)))
        workspace = _workspace("attn", q.device, need, zero=False)
    args = (ctypes.byref(d), B, N, Hq, _ptr(ctx_lens), int(max_ctx), _ptr(q), _dtype_code(q), _ptr(parent),
            float(sm_scale))
    tail = (_ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device))
    if t is not None:
        rc = lib.sv_verify_attn_tuned(*args, int(window), _tref(t), *tail)
        _check_ws(rc, "sv_verify_attn_tuned", "attn", q.device, default_ws)
    elif window:
        rc = lib.sv_verify_attn_window(*args, int(window), *tail)
        _check_ws(rc, "sv_verify_attn_window", "attn", q.device, default_ws)
    else:
        rc = lib.sv_verify_attn(*args, *tail)
        _check_ws(rc, "sv_verify_attn", "attn", q.device, default_ws)
    return out, lse


def verify_attn_noalloc(kv: KVCache, q: torch.Tensor, ctx_lens: torch.Tensor, parent: torch.Tensor,
                        max_ctx: int, out: torch.Tensor, lse: Optional[torch.Tensor] = None, sm_scale: float = 0.0,
                        layer: int = 0, window: int = 0):
    """verify_attn through sv_verify_attn_noalloc: no workspace (the library's
    static per-GPU buffer of NOALLOC_SCRATCH_BYTES holds the split partials;
    calls that overlap on one GPU race), and the caller passes the outputs, so
    nothing is allocated."""
    if q.dim() != 4 or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q must be a contiguous [B, N, Hq, D] device tensor")
    B, N, Hq, D = q.shape
    _i32(ctx_lens, "ctx_lens")
    _i32(parent, "parent")
    if out is None or out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped like q")
    d = kv.desc(layer)
    rc = lib.sv_verify_attn_noalloc(ctypes.byref(d), B, N, Hq, _ptr(ctx_lens), int(max_ctx), _ptr(q),
                                    _dtype_code(q), _ptr(parent), float(sm_scale), int(window), _ptr(out), _ptr(lse),
                                    _stream(q.device))
    _check(rc, "sv_verify_attn_noalloc")
    return out, lse


def greedy_accept_workspace_size(batch: int, n_nodes: int, vocab: int) -> int:
    return int(lib.sv_greedy_accept_workspace_size(batch, n_nodes, vocab))


def greedy_accept(logits: torch.Tensor, draft_ids: torch.Tensor, parent: torch.Tensor,
                  want_argmax: bool = True, workspace: Optional[torch.Tensor] = None, outputs=None,
                  tuning: Optional[dict] = None):
    """Greedy acceptance.  ``logits`` ``[B, N, V]`` fp32/bf16.

    Returns ``(accept_len [B], path [B, N], tokens [B, N], argmax [B, N] or None)``.
    """
    if logits.dim() != 3 or not logits.is_contiguous() or not logits.is_cuda:
        raise ValueError("logits must be a contiguous [B, N, V] device tensor")
    B, N, V = logits.shape
    _i32(draft_ids, "draft_ids")
    _i32(parent, "parent")
    dev = logits.device
    if outputs is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
        tok = torch.empty((B, N), dtype=torch.int32, device=dev)
        am = torch.empty((B, N), dtype=torch.int32, device=dev) if want_argmax else None
    else:
        acc, path, tok, am = outputs
    need = int(lib.sv_greedy_accept_workspace_size(B, N, V))
    default_ws = workspace is None
    if default_ws:
        workspace = _workspace("accept", dev, need, zero=True)
    t = _tuning(tuning)
    if t is not None:
        rc = lib.sv_greedy_accept_tuned(B, N, V, _ptr(logits), _dtype_code(logits), _ptr(draft_ids), _ptr(parent),
                                        _ptr(acc), _ptr(path), _ptr(tok), _ptr(am), _tref(t), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(dev))
        _check_ws(rc, "sv_greedy_accept_tuned", "accept", dev, default_ws)
        return acc, path, tok, am
    rc = lib.sv_greedy_accept(B, N, V, _ptr(logits), _dtype_code(logits), _ptr(draft_ids), _ptr(parent),
                              _ptr(acc), _ptr(path), _ptr(tok), _ptr(am), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(dev))
    _check_ws(rc, "sv_greedy_accept", "accept", dev, default_ws)
    return acc, path, tok, am


def sample_accept(logits: torch.Tensor, gumbel: torch.Tensor, temperature: float, draft_ids: torch.Tensor,
                  parent: torch.Tensor, want_samples: bool = True, workspace: Optional[torch.Tensor] = None,
                  outputs=None, top_k: int = 0):
    """Stochastic verification at ``temperature`` with the caller's standard
    Gumbel noise ``gumbel`` (float32, the shape of ``logits``); ``top_k`` > 0
    samples among each row's top-k tokens.

    Returns ``(accept_len [B], path [B, N], tokens [B, N], samples [B, N] or None)``.
    """
    if logits.dim() != 3 or not logits.is_contiguous() or not logits.is_cuda:
        raise ValueError("logits must be a contiguous [B, N, V] device tensor")
    if gumbel.shape != logits.shape or gumbel.dtype != torch.float32 or not gumbel.is_contiguous():
        raise ValueError("gumbel must be a contiguous float32 tensor shaped like logits")
    B, N, V = logits.shape
    _i32(draft_ids, "draft_ids")
    _i32(parent, "parent")
    dev = logits.device
    if outputs is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
        tok = torch.empty((B, N), dtype=torch.int32, device=dev)
        ys = torch.empty((B, N), dtype=torch.int32, device=dev) if want_samples else None
    else:
        acc, path, tok, ys = outputs
    need = int(lib.sv_greedy_accept_workspace_size(B, N, V))
    default_ws = workspace is None
    if default_ws:
        workspace = _workspace("accept", dev, need, zero=True)
    if top_k:
        rc = lib.sv_sample_accept_topk(B, N, V, _ptr(logits), _dtype_code(logits), _ptr(gumbel), float(temperature),
                                       int(top_k), _ptr(draft_ids), _ptr(parent), _ptr(acc), _ptr(path), _ptr(tok),
                                       _ptr(ys), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(dev))
        _check_ws(rc, "sv_sample_accept_topk", "accept", dev, default_ws)
        return acc, path, tok, ys
    rc = lib.sv_sample_accept(B, N, V, _ptr(logits), _dtype_code(logits), _ptr(gumbel), float(temperature),
                              _ptr(draft_ids), _ptr(parent), _ptr(acc), _ptr(path), _ptr(tok), _ptr(ys),
                              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check_ws(rc, "sv_sample_accept", "accept", dev, default_ws)
    return acc, path, tok, ys


def kv_compact(kv: KVCache, ctx_lens: torch.Tensor, max_ctx: int, path: torch.Tensor,
               accept_len: torch.Tensor, n_layers: Optional[int] = None,
               new_lens: Optional[torch.Tensor] = None) -> torch.Tensor:
    """In-place compaction of the accepted rows (every layer of ``kv``)."""
    _i32(ctx_lens, "ctx_lens")
    _i32(path, "path")
    _i32(accept_len, "accept_len")
    B, N = path.shape
    if new_lens is None:
        new_lens = torch.empty(B, dtype=torch.int32, device=path.device)
    d = kv.desc(0)
    L = kv.n_layers if n_layers is None else n_layers
    rc = lib.sv_kv_compact(ctypes.byref(d), L, B, N, _ptr(ctx_lens), int(max_ctx), _ptr(path),
                           _ptr(accept_len), _ptr(new_lens), _stream(path.device))
    _check(rc, "sv_kv_compact")
    return new_lens


def greedy_accept_compact(logits: torch.Tensor, draft_ids: torch.Tensor, parent: torch.Tensor, kv: KVCache,
                          ctx_lens: torch.Tensor, max_ctx: int, want_argmax: bool = True,
                          workspace: Optional[torch.Tensor] = None, outputs=None, n_layers: Optional[int] = None,
                          new_lens: Optional[torch.Tensor] = None):
    """``greedy_accept`` then ``kv_compact`` in one launch.

    Returns ``(accept_len, path, tokens, argmax or None, new_lens)``.
    """
    if logits.dim() != 3 or not logits.is_contiguous() or not logits.is_cuda:
        raise ValueError("logits must be a contiguous [B, N, V] device tensor")
    B, N, V = logits.shape
    _i32(draft_ids, "draft_ids")
    _i32(parent, "parent")
    _i32(ctx_lens, "ctx_lens")
    dev = logits.device
    if outputs is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
        tok = torch.empty((B, N), dtype=torch.int32, device=dev)
        am = torch.empty((B, N), dtype=torch.int32, device=dev) if want_argmax else None
    else:
        acc, path, tok, am = outputs
    if new_lens is None:
        new_lens = torch.empty(B, dtype=torch.int32, device=dev)
    need = int(lib.sv_greedy_accept_workspace_size(B, N, V))
    default_ws = workspace is None
    if default_ws:
        workspace = _workspace("accept", dev, need, zero=True)
    d = kv.desc(0)
    L = kv.n_layers if n_layers is None else n_layers
    rc = lib.sv_greedy_accept_compact(B, N, V, _ptr(logits), _dtype_code(logits), _ptr(draft_ids), _ptr(parent),
                                      _ptr(acc), _ptr(path), _ptr(tok), _ptr(am), ctypes.byref(d), L,
                                      _ptr(ctx_lens), int(max_ctx), _ptr(new_lens), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(dev))
    _check_ws(rc, "sv_greedy_accept_compact", "accept", dev, default_ws)
    return acc, path, tok, am, new_lens


def kv_append(kv: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, ctx_lens: torch.Tensor, max_ctx: int) -> None:
    """Write the verify block's rows ``[B, n, Hkv, D]`` (fp32 or bf16) into layer 0
    of ``kv`` at positions ctx .. ctx + n - 1 (quantised for a 4-bit cache)."""
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if t.dim() != 4 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous [B, n, Hkv, D] device tensor")
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new differ in shape or dtype")
    _i32(ctx_lens, "ctx_lens")
    B, n, H, D = k_new.shape
    d = kv.desc(0)
    rc = lib.sv_kv_append(ctypes.byref(d), B, n, _ptr(ctx_lens), int(max_ctx), _ptr(k_new), _ptr(v_new),
                          _dtype_code(k_new), _stream(k_new.device))
    _check(rc, "sv_kv_append")


def _dev(t: torch.Tensor, name: str, dim: int) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != dim:
        raise ValueError(f"{name} must be a {dim}-d device tensor")


def _state_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.float16:
        return SV_F16
    raise TypeError(f"per-node states must be float32 or float16, not {t.dtype}")


def ssm_conv_tree(x: torch.Tensor, conv_state: torch.Tensor, weight: torch.Tensor,
                  bias: Optional[torch.Tensor] = None, parent: Optional[torch.Tensor] = None,
                  activation: str = "silu", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal depthwise conv of the verify block ``x [B, N, C]`` with each node's
    window along its parent chain (then ``conv_state [B, K-1, C]``); ``weight
    [C, K]`` fp32, tap K-1 on the node itself; SiLU when ``activation == "silu"``."""
    _dev(x, "x", 3)
    _dev(conv_state, "conv_state", 3)
    _dev(weight, "weight", 2)
    B, N, C = x.shape
    K = weight.shape[1]
    for t, name in ((x, "x"), (conv_state, "conv_state"), (weight, "weight")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if conv_state.shape != (B, K - 1, C) or conv_state.dtype != x.dtype:
        raise ValueError("conv_state must be [B, K-1, C] in x's dtype")
    if weight.dtype != torch.float32 or weight.shape[0] != C:
        raise ValueError("weight must be float32 [C, K]")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (C,) or not bias.is_contiguous()):
        raise ValueError("bias must be float32 [C]")
    if parent is not None:
        _i32(parent, "parent")
    if activation not in ("silu", "none"):
        raise ValueError("activation is 'silu' or 'none'")
    if out is None:
        out = torch.empty_like(x)
    rc = lib.sv_ssm_conv_tree(B, N, C, K, _ptr(x), _ptr(conv_state), _dtype_code(x), _ptr(weight), _ptr(bias),
                              _ptr(parent), 1 if activation == "silu" else 0, _ptr(out), _stream(x.device))
    _check(rc, "sv_ssm_conv_tree")
    return out


def _token_stride(t: torch.Tensor, name: str) -> int:
    """Row stride of a [B, N, H, D] view whose (H, D) block is packed."""
    _dev(t, name, 4)
    B, N, H, D = t.shape
    s = t.stride()
    if s[3] != 1 or s[2] != D or (B > 1 and s[0] != N * s[1]):
        raise ValueError(f"{name} must be [B, N, H, D] with packed heads and a uniform token stride")
    return s[1]


def tree_schedule(parent: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The visiting order words of every tree in ``parent [B, N]`` (int32 ``[B, 64]``),
    shared by the recurrent layers of one verify step."""
    _i32(parent, "parent")
    B, N = parent.shape
    if out is None:
        out = torch.empty((B, 64), dtype=torch.int32, device=parent.device)
    rc = lib.sv_tree_schedule(B, N, _ptr(parent), _ptr(out), _stream(parent.device))
    _check(rc, "sv_tree_schedule")
    return out


def gated_delta_net_tree(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                         state: torch.Tensor, parent: Optional[torch.Tensor] = None, scale: float = 0.0,
                         state_dtype: torch.dtype = torch.float16, out: Optional[torch.Tensor] = None,
                         state_nodes: Optional[torch.Tensor] = None, schedule: Optional[torch.Tensor] = None):
    """Gated delta rule over the verify tree: returns ``(out [B, N, Hv, Dv],
    state_nodes [B, N, Hv, Dv, Dk])``.  ``q``/``k`` ``[B, N, Hk, Dk]`` and ``v``
    ``[B, N, Hv, Dv]`` (fp32 or bf16; views into one packed buffer are fine),
    ``g``/``beta`` fp32 ``[B, N, Hv]``, ``state`` fp32 ``[B, Hv, Dv, Dk]``."""
    sq, sk, sv_ = _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v")
    if sq != sk or q.shape != k.shape or q.dtype != k.dtype or v.dtype != q.dtype:
        raise ValueError("q and k must share shape, token stride and dtype (v the dtype)")
    B, N, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    if v.shape[:2] != (B, N):
        raise ValueError("v must be [B, N, Hv, Dv]")
    for t, name in ((g, "g"), (beta, "beta")):
        if t.dtype != torch.float32 or t.shape != (B, N, Hv) or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous float32 [B, N, Hv] device tensor")
    if state.dtype != torch.float32 or state.shape != (B, Hv, Dv, Dk) or not state.is_contiguous():
        raise ValueError("state must be a contiguous float32 [B, Hv, Dv, Dk] tensor")
    if parent is not None:
        _i32(parent, "parent")
    if schedule is not None:
        _i32(schedule, "schedule")
        if schedule.shape != (B, 64):
            raise ValueError("schedule must be int32 [B, 64] from tree_schedule")
    if out is None:
        out = torch.empty((B, N, Hv, Dv), dtype=q.dtype, device=q.device)
    if state_nodes is None:
        state_nodes = torch.empty((B, N, Hv, Dv, Dk), dtype=state_dtype, device=q.device)
    if state_nodes.shape != (B, N, Hv, Dv, Dk) or not state_nodes.is_contiguous():
        raise ValueError("state_nodes must be a contiguous [B, N, Hv, Dv, Dk] tensor")
    rc = lib.sv_gated_delta_net_tree(B, N, Hk, Hv, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), sq, sv_, _dtype_code(q),
                                     _ptr(g), _ptr(beta), _ptr(state), _ptr(parent), _ptr(schedule), float(scale),
                                     _ptr(out),
                                     _ptr(state_nodes), _state_code(state_nodes), _stream(q.device))
    _check(rc, "sv_gated_delta_net_tree")
    return out, state_nodes


def recurrent_commit(state_nodes: torch.Tensor, state: torch.Tensor, x: torch.Tensor, conv_state: torch.Tensor,
                     path: torch.Tensor, accept_len: torch.Tensor) -> None:
    """In place: ``state[b] <- state_nodes[b, path[b, a]]`` and ``conv_state[b]`` <-
    the last K-1 of (conv_state[b], x[b, path[b, 0..a]]), a = accept_len[b]."""
    _dev(state_nodes, "state_nodes", 5)
    B, N, Hv, Dv, Dk = state_nodes.shape
    if state.dtype != torch.float32 or state.shape != (B, Hv, Dv, Dk) or not state.is_contiguous():
        raise ValueError("state must be a contiguous float32 [B, Hv, Dv, Dk] tensor")
    _dev(x, "x", 3)
    _dev(conv_state, "conv_state", 3)
    C = x.shape[2]
    if x.shape[:2] != (B, N) or conv_state.shape[0] != B or conv_state.shape[2] != C or conv_state.dtype != x.dtype:
        raise ValueError("x must be [B, N, C] and conv_state [B, K-1, C] in one dtype")
    for t, name in ((state_nodes, "state_nodes"), (x, "x"), (conv_state, "conv_state")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _i32(path, "path")
    _i32(accept_len, "accept_len")
    rc = lib.sv_recurrent_commit(B, N, Hv, Dk, Dv, _ptr(state_nodes), _state_code(state_nodes), _ptr(state), C,
                                 conv_state.shape[1] + 1, _ptr(x), _ptr(conv_state), _dtype_code(x), _ptr(path),
                                 _ptr(accept_len), _stream(x.device))
    _check(rc, "sv_recurrent_commit")


def check_device_errors(device=None) -> int:
    """The precondition bits (SV_DEVERR_*) recorded on ``device`` since the
    previous check, then cleared; waits for the device's current stream.
    Always 0 with the release library."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        rc = int(lib.sv_check_device_errors(_stream(dev)))
    if rc < 0:
        raise SVError(rc, "sv_check_device_errors")
    return rc
