"""Pins of the oracle's cache write (the verify block's K/V rows into the cache,
4-bit quantisation at write time) against hand-worked blocks, library routines,
an independently written quantiser and properties of the format."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.append import bf16_round, kv_append, q4_quantise

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q4_write_blocks.json")


def test_hand_worked_blocks():
    g = json.load(open(GOLDEN))
    x = np.array([b["x"] for b in g["blocks"]], dtype=np.float32).reshape(1, 96)
    codes, scales = q4_quantise(x)
    assert scales[0].tolist() == [b["scale_bits"] for b in g["blocks"]]
    assert codes[0].tolist() == sum((b["bytes"] for b in g["blocks"]), [])


def test_bf16_rounding_hand_worked_and_library():
    g = json.load(open(GOLDEN))["bf16_rounding"]
    u = np.array([p[0] for p in g["pairs"]], dtype=np.uint32)
    assert bf16_round(u.view(np.float32)).tolist() == [p[1] for p in g["pairs"]]
    # torch's fp32 -> bf16 conversion rounds to nearest even as well (finite values)
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ties = (x.view(np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_round(x), ref)


def test_quantiser_agrees_with_independent_harness_quantiser():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((6, 256)) * rng.uniform(0.01, 50, (6, 1))).astype(np.float32)
    x[2, 32:64] = 0.0                                     # a zero block
    x[3, :32] = np.float32(0.5) * np.arange(-16, 16)      # ties of x / d
    c1, s1 = q4_quantise(x)
    c2, s2 = workloads.q4_encode(x)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)


def test_quantisation_error_bound_and_code_range():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((8, 128)) * rng.uniform(1e-3, 100, (8, 1))).astype(np.float32)
    codes, scales = q4_quantise(x)
    back = oracle.q4_decode(codes, scales)
    d = np.repeat(oracle.widen_fp16(scales), 32, axis=-1)
    # |x / d| <= 7 * (1 + 2^-11) after the half rounding of d, so no value is
    # clamped beyond half a step: the error is at most d/2 (+ the division's rounding)
    assert np.all(np.abs(back - x.astype(np.float64)) <= d * (0.5 + 1e-6))
    lo = codes & 0x0F
    hi = codes >> 4
    n = np.concatenate([lo, hi], axis=-1)
    assert n.min() >= 1 and n.max() <= 15                # max|x| / d rounds to 7 at most


def test_kv_append_contiguous_and_paged():
    rng = np.random.default_rng(7)
    B, H, D, n, cap = 2, 3, 64, 4, 20
    k = rng.integers(0, 2**16, (B, H, cap, D), dtype=np.uint16)
    v = rng.integers(0, 2**16, (B, H, cap, D), dtype=np.uint16)
    nk = rng.standard_normal((B, n, H, D)).astype(np.float32)
    nv = rng.standard_normal((B, n, H, D)).astype(np.float32)
    ctx = np.array([3, 40])                               # 40 clamps to max_ctx = 16
    out = kv_append([k, v], nk, nv, ctx_lens=ctx, dtype="bf16", src_dtype="f32", max_ctx=16)
    for b, c in [(0, 3), (1, 16)]:
        for h in range(H):
            np.testing.assert_array_equal(out[0][b, h, c:c + n], bf16_round(nk[b, :, h]))
            np.testing.assert_array_equal(out[1][b, h, c:c + n], bf16_round(nv[b, :, h]))
            keep = np.ones(cap, bool)
            keep[c:c + n] = False
            np.testing.assert_array_equal(out[0][b, h, keep], k[b, h, keep])
    # paged, 4-bit, bf16 source rows: page 1 of sequence 0 is outside the pool
    ps, pages = 4, 6
    kc = rng.integers(0, 256, (pages, H, ps, D // 2), dtype=np.uint8)
    vc = rng.integers(0, 256, (pages, H, ps, D // 2), dtype=np.uint8)
    ks = rng.integers(0, 2**15, (pages, H, ps, D // 32), dtype=np.uint16)
    vs = rng.integers(0, 2**15, (pages, H, ps, D // 32), dtype=np.uint16)
    pt = np.array([[2, 9, 4], [5, 0, 1]])
    nkb = workloads.bf16_bits(nk)
    nvb = workloads.bf16_bits(nv)
    out = kv_append([kc, vc, ks, vs], nkb, nvb, ctx_lens=np.array([2, 5]), dtype="q4", src_dtype="bf16",
                    page_table=pt, page_size=ps)
    exp_c, exp_s = q4_quantise(oracle.widen_bf16(nkb).astype(np.float32))
    # sequence 0 rows 0, 1 -> positions 2, 3 (page 2); rows 2, 3 -> page id 9: skipped
    np.testing.assert_array_equal(out[0][2, :, 2:4], np.transpose(exp_c[0, 0:2], (1, 0, 2)))
    np.testing.assert_array_equal(out[2][2, :, 2:4], np.transpose(exp_s[0, 0:2], (1, 0, 2)))
    # sequence 1 rows 0..2 -> positions 5..7 (page 0, slots 1..3), row 3 -> position 8 (page 1, slot 0)
    np.testing.assert_array_equal(out[0][0, :, 1:4], np.transpose(exp_c[1, 0:3], (1, 0, 2)))
    np.testing.assert_array_equal(out[0][1, :, 0], exp_c[1, 3])
    untouched = [p for p in range(pages) if p not in (0, 1, 2)]
    for p in untouched:
        np.testing.assert_array_equal(out[0][p], kc[p])
        np.testing.assert_array_equal(out[3][p], vs[p])


def test_kv_append_f32_cache_from_bf16_is_exact_widening():
    rng = np.random.default_rng(8)
    k = np.zeros((1, 1, 8, 32), np.float32)
    nk = workloads.bf16_bits(rng.standard_normal((1, 2, 1, 32)).astype(np.float32))
    out = kv_append([k, k.copy()], nk, nk, ctx_lens=[5], dtype="f32", src_dtype="bf16")
    np.testing.assert_array_equal(out[0][0, 0, 5:7], oracle.widen_bf16(nk[0, :, 0]).astype(np.float32))
